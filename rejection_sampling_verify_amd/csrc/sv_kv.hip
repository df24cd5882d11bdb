// sv_kv.hip — KV-cache rollback after verification ("7.6 Speculative
// Decoding: Draft Models, Medusa, EAGLE & Lookahead", "KV-Cache Reuse and
// Rollback"): every layer's cache keeps the committed prefix and the accepted
// path's entries, gathered along the sequence dimension; a chain's path is the
// identity, so a chain step only shortens the cache.
//
// One wavefront per (layer, sequence, head) slab of [positions, head_dim]. The
// lanes check the path together, then move its rows as 16-byte vectors, a
// chunk of rows at a time, every vector of a chunk read before any is written:
// node k comes from node p_k >= k and the path increases, so the sources of
// later chunks (rows p_j > p_k >= k) lie past every row an earlier chunk wrote,
// and within a chunk the barrier orders the reads before the writes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/spec_verify.h"
#include "sv_internal.h"

namespace sv {
namespace {

typedef uint32_t kv_u32x4 __attribute__((ext_vector_type(4)));
constexpr int kKvThreads = 64;      // one wavefront per slab
constexpr int kKvPerLane = 4;       // 16-byte vectors a lane holds per chunk (K and V each)
constexpr int kKvMaxPath = 1024;    // path entries staged in LDS (a tree has at most SV_MAX_TREE_NODES nodes)
constexpr int kKvMaxRowBytes = 16384;

struct KvArgs {
  uint8_t* k;  // [L, B, H, S, D] elements of elem bytes
  uint8_t* v;  // same layout, or NULL
  int32_t L, B, H, S;
  int32_t vpr;              // 16-byte vectors per row (D * elem / 16)
  const int32_t* root;      // [B]
  const int32_t* path;      // [B, P]
  int32_t P;
  const int32_t* path_len;  // [B]
  int32_t* cache_len;       // [B] out
};

__global__ __launch_bounds__(kKvThreads) void kv_rollback_kernel(KvArgs a) {
  extern __shared__ int32_t s_path[];  // [P]
  const int64_t slab = blockIdx.x;     // (l, b, h), h fastest
  const int h = (int)(slab % a.H);
  const int b = (int)((slab / a.H) % a.B);
  const int l = (int)(slab / ((int64_t)a.H * a.B));
  const int lane = (int)threadIdx.x;
  const int n = a.path_len[b];
  const int r = a.root[b];
  // The oracle's validity rule: root first, strictly increasing nodes, every
  // position inside the cache (which also keeps every node >= 0).
  int bad = !(n >= 1 && n <= a.P && r >= 0);
  if (!bad)
    for (int k = lane; k < n; k += kKvThreads) s_path[k] = a.path[(int64_t)b * a.P + k];
  __syncthreads();
  if (!bad)
    for (int k = lane; k < n; k += kKvThreads) {
      const int p = s_path[k];
      bad |= !((k == 0 ? p == 0 : p > s_path[k - 1]) && (int64_t)r + p < a.S);
    }
  bad = __syncthreads_or(bad);
  if (lane == 0 && l == 0 && h == 0) a.cache_len[b] = bad ? -1 : r + n;
  if (bad) return;
  const int vpr = a.vpr;
  const int64_t row_bytes = (int64_t)vpr * 16;
  const int64_t slab_off = slab * a.S * row_bytes;
  const int items = n * vpr;  // (node, vector) pairs, vector fastest
  for (int i0 = 0; i0 < items; i0 += kKvThreads * kKvPerLane) {
    kv_u32x4 qk[kKvPerLane], qv[kKvPerLane];
#pragma unroll
    for (int j = 0; j < kKvPerLane; ++j) {
      const int i = i0 + j * kKvThreads + lane;
      const int k = i / vpr;
      if (i < items && s_path[k] != k) {
        const int64_t src = slab_off + (int64_t)(r + s_path[k]) * row_bytes + (int64_t)(i - k * vpr) * 16;
        qk[j] = *(const kv_u32x4*)(a.k + src);
        if (a.v) qv[j] = *(const kv_u32x4*)(a.v + src);
      }
    }
    __syncthreads();  // the whole chunk is read before any of it is written
#pragma unroll
    for (int j = 0; j < kKvPerLane; ++j) {
      const int i = i0 + j * kKvThreads + lane;
      const int k = i / vpr;
      if (i < items && s_path[k] != k) {
        const int64_t dst = slab_off + (int64_t)(r + k) * row_bytes + (int64_t)(i - k * vpr) * 16;
        *(kv_u32x4*)(a.k + dst) = qk[j];
        if (a.v) *(kv_u32x4*)(a.v + dst) = qv[j];
      }
    }
    __syncthreads();
  }
}

}  // namespace
}  // namespace sv

extern "C" {

sv_status_t sv_kv_rollback(void* k_cache, void* v_cache, int32_t elem_bytes, int32_t L, int32_t B, int32_t H,
                           int32_t S, int32_t D, const int32_t* root_pos, const int32_t* path, int32_t P,
                           const int32_t* path_len, int32_t* cache_len, void* stream) {
  if (!k_cache || !root_pos || !path || !path_len || !cache_len) return SV_ERR_NULL_ARG;
  if (L < 0 || B < 0 || H < 0 || S < 1 || D < 1 || P < 1 || P > sv::kKvMaxPath) return SV_ERR_BAD_SHAPE;
  if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4) return SV_ERR_BAD_DTYPE;
  // Rows move as 16-byte vectors: a row is a whole number of them and the
  // caches are 16-byte aligned.
  const int64_t row_bytes = (int64_t)D * elem_bytes;
  if (row_bytes % 16 != 0 || row_bytes > sv::kKvMaxRowBytes) return SV_ERR_BAD_SHAPE;
  if ((uintptr_t)k_cache % 16 != 0 || (uintptr_t)v_cache % 16 != 0) return SV_ERR_BAD_ARG;
  const int64_t slabs = (int64_t)L * B * H;
  if (slabs >= (1ll << 31)) return SV_ERR_BAD_SHAPE;
  if (slabs == 0) return SV_OK;
  sv::KvArgs a;
  a.k = (uint8_t*)k_cache;
  a.v = (uint8_t*)v_cache;
  a.L = L;
  a.B = B;
  a.H = H;
  a.S = S;
  a.vpr = (int32_t)(row_bytes / 16);
  a.root = root_pos;
  a.path = path;
  a.P = P;
  a.path_len = path_len;
  a.cache_len = cache_len;
  hipLaunchKernelGGL(sv::kv_rollback_kernel, dim3((unsigned)slabs), dim3(sv::kKvThreads), P * sizeof(int32_t),
                     (hipStream_t)stream, a);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}

}  // extern "C"
