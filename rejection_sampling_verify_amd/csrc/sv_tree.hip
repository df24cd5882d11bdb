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
// One workgroup per (sequence, node, chunk) computes a partial argmax; the
// last one of a sequence merges them in fixed order and walks the tree. No
// workgroup waits on another; partials travel through exchange operations.
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
  uint32_t last;
  int32_t bad_tree, bad_tok;
  int32_t g[kMaxTreeNodes];
  int32_t par[kMaxTreeNodes];
  int32_t dep[kMaxTreeNodes];
  int32_t tok[kMaxTreeNodes];
  uint8_t alive[kMaxTreeNodes];
};

__device__ void tree_decide(const TreeArgs& a, int b, TreeSmem& sm) {
  const int N = a.N, C = a.nchunks, tid = threadIdx.x;
  const int32_t* tok = a.tokens + (int64_t)b * N;
  if (tid == 0) {
    sm.bad_tree = 0;
    sm.bad_tok = 0;
  }
  __syncthreads();
  // Stage the tree and merge each node's argmax over its chunks, in order.
  for (int node = tid; node < N; node += kThreads) {
    ArgMax m;
    m.v = -INFINITY;
    m.i = -1;
    TreePartial* pp = a.part + ((int64_t)b * N + node) * C;
#pragma unroll 4
    for (int c = 0; c < C; ++c) {
      ArgMax o;
      o.v = xget(&pp[c].v);
      o.i = xget(&pp[c].i);
      m = argmax_merge(m, o);
    }
    sm.g[node] = m.i;
    sm.par[node] = a.parents[node];
    sm.dep[node] = a.depth[node];
    sm.tok[node] = tok[node];
  }
  __syncthreads();
  // The tree must be in parent-before-child order with consistent depths.
  for (int i = tid; i < N; i += kThreads) {
    bool ok;
    if (i == 0) {
      ok = (sm.par[0] == -1) && (sm.dep[0] == 0);
    } else {
      const int p = sm.par[i];
      ok = (p >= 0) && (p < i) && (sm.dep[i] == sm.dep[p] + 1) && (sm.dep[i] <= a.max_depth);
      if (sm.tok[i] < 0 || sm.tok[i] >= a.V) atomicOr(&sm.bad_tok, 1);
    }
    if (!ok) atomicOr(&sm.bad_tree, 1);
  }
  __syncthreads();
  if (tid == 0) {
    int32_t* path = a.out_path + (int64_t)b * (a.max_depth + 1);
    for (int k = 0; k <= a.max_depth; ++k) path[k] = -1;
    if (sm.bad_tree) {
      a.out_path_len[b] = -3;
      a.out_bonus[b] = -1;
    } else if (sm.bad_tok) {
      a.out_path_len[b] = -1;
      a.out_bonus[b] = -1;
    } else {
      // Survival in index order: a parent precedes its children.
      sm.alive[0] = 1;
      int best = 0;
      for (int c = 1; c < N; ++c) {
        const int p = sm.par[c];
        const uint8_t alive = (sm.alive[p] && sm.tok[c] == sm.g[p]) ? 1 : 0;
        sm.alive[c] = alive;
        if (alive && sm.dep[c] > sm.dep[best]) best = c;
      }
      const int len = sm.dep[best] + 1;
      for (int c = best, k = len - 1; c != -1; c = sm.par[c], --k) path[k] = c;
      a.out_path_len[b] = len;
      a.out_bonus[b] = sm.g[best];
    }
  }
  // Return the scratch of b to zero.
  uint32_t* words = (uint32_t*)(a.part + (int64_t)b * N * C);
  for (int k = tid; k < N * C * 2; k += kThreads) xput(&words[k], 0u);
  if (tid == 0) xput(&a.arrive[b], 0u);
}

template <bool BF16, bool VEC>
__global__ __launch_bounds__(kThreads) void tree_kernel(TreeArgs a) {
  __shared__ TreeSmem sm;
  const int per_seq = a.N * a.nchunks;
  const int b = blockIdx.x / per_seq;
  const int r = blockIdx.x % per_seq;
  const int node = r / a.nchunks;
  const int c = r % a.nchunks;
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
    TreePartial* p = a.part + ((int64_t)b * a.N + node) * a.nchunks + c;
    xput(&p->v, t.v);
    xput(&p->i, t.i);
    wait_vmem();
    const uint32_t old = atomicAdd(&a.arrive[b], 1u);
    sm.last = (old == (uint32_t)per_seq - 1u) ? 1u : 0u;
  }
  __syncthreads();
  if (sm.last) tree_decide(a, b, sm);
}

template <bool BF16, bool VEC>
hipError_t launch_tree_t(const TreeArgs& a, hipStream_t stream) {
  const long long grid = (long long)a.B * a.N * a.nchunks;
  hipLaunchKernelGGL((tree_kernel<BF16, VEC>), dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_tree(const TreeArgs& a, bool bf16, bool vec, hipStream_t stream) {
  if (bf16) return vec ? launch_tree_t<true, true>(a, stream) : launch_tree_t<true, false>(a, stream);
  return vec ? launch_tree_t<false, true>(a, stream) : launch_tree_t<false, false>(a, stream);
}

}  // namespace sv
