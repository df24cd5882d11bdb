// sv_kv.hip — KV-cache rollback after verification ("7.6 Speculative
// Decoding: Draft Models, Medusa, EAGLE & Lookahead", "KV-Cache Reuse and
// Rollback"): every layer's cache keeps the committed prefix and the accepted
// path's entries, gathered along the sequence dimension; a chain's path is the
// identity, so a chain step only shortens the cache.
//
// One workgroup per (layer, sequence), covering every head: the lanes check the
// path together, then move its rows as 16-byte vectors, a chunk of (head, node,
// vector) items at a time, every item of a chunk read before any is written.
// Within one head node k comes from node p_k >= k and the path increases, so
// the sources of later chunks (rows p_j > p_k >= k) lie past every row an
// earlier chunk wrote there, and inside a chunk the barrier orders the reads
// before the writes; heads are disjoint slabs.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/spec_verify.h"

namespace sv {
namespace {

typedef uint32_t kv_u32x4 __attribute__((ext_vector_type(4)));
constexpr int kKvThreads = 256;
constexpr int kKvPerLane = 4;       // 16-byte vectors a lane holds per chunk (K and V each)
constexpr int kKvMaxPath = 1024;    // path entries staged in LDS (a tree has at most SV_MAX_TREE_NODES nodes)
constexpr int kKvMaxRowBytes = 16384;

struct KvArgs {
  uint8_t* k;  // [L, B, H, S, D] elements of elem bytes (stacked layers)
  uint8_t* v;  // same layout, or NULL
  const uint64_t* k_layers;  // or: device array of L pointers to [B, H, S, D] caches
  const uint64_t* v_layers;  // same, or NULL
  int32_t B, H, S;
  int32_t vpr;              // 16-byte vectors per row (D * elem / 16)
  const int32_t* root;      // [B]
  const int32_t* path;      // [B, P]
  int32_t P;
  const int32_t* path_len;  // [B]
  int32_t* cache_len;       // [B] out
};

// LAYERS: each layer's cache is its own allocation, found in k_layers /
// v_layers; else the layers are stacked in k / v.
template <bool LAYERS>
__global__ __launch_bounds__(kKvThreads) void kv_rollback_kernel(KvArgs a) {
  extern __shared__ int32_t s_path[];  // [P]
  const int64_t lb = blockIdx.x;       // (l, b), b fastest
  const int b = (int)(lb % a.B);
  const int l = (int)(lb / a.B);
  const int tid = (int)threadIdx.x;
  // The whole path row is staged whatever its length, so that its loads and
  // those of the length and the root share one trip to memory.
  for (int k = tid; k < a.P; k += kKvThreads) s_path[k] = a.path[(int64_t)b * a.P + k];
  const int n = a.path_len[b];
  const int r = a.root[b];
  __syncthreads();
  // The oracle's validity rule: root first, strictly increasing nodes, every
  // position inside the cache (which also keeps every node >= 0).
  int bad = !(n >= 1 && n <= a.P && r >= 0);
  if (!bad)
    for (int k = tid; k < n; k += kKvThreads) {
      const int p = s_path[k];
      bad |= !((k == 0 ? p == 0 : p > s_path[k - 1]) && (int64_t)r + p < a.S);
    }
  bad = __syncthreads_or(bad);
  if (tid == 0 && l == 0) a.cache_len[b] = bad ? -1 : r + n;
  if (bad) return;
  const int vpr = a.vpr;
  const int per_head = n * vpr;
  const int items = a.H * per_head;  // (head, node, vector), vector fastest; < 2^31 (checked on the host)
  const int64_t row_bytes = (int64_t)vpr * 16;
  const int64_t head_bytes = (int64_t)a.S * row_bytes;
  uint8_t* kbase = a.k;
  uint8_t* vbase = a.v;
  int64_t lb_off = lb * a.H * head_bytes + (int64_t)r * row_bytes;
  if (LAYERS) {
    kbase = (uint8_t*)a.k_layers[l];
    vbase = a.v_layers ? (uint8_t*)a.v_layers[l] : nullptr;
    lb_off = (int64_t)b * a.H * head_bytes + (int64_t)r * row_bytes;
  }
  for (int i0 = 0; i0 < items; i0 += kKvThreads * kKvPerLane) {
    kv_u32x4 qk[kKvPerLane], qv[kKvPerLane];
    int64_t dst[kKvPerLane];
    bool act[kKvPerLane];
#pragma unroll
    for (int j = 0; j < kKvPerLane; ++j) {
      const int i = i0 + j * kKvThreads + tid;
      act[j] = false;
      if (i < items) {
        const int h = i / per_head;
        const int rem = i - h * per_head;
        const int k = rem / vpr;
        const int64_t base = lb_off + h * head_bytes + (int64_t)(rem - k * vpr) * 16;
        const int p = s_path[k];
        act[j] = p != k;
        dst[j] = base + (int64_t)k * row_bytes;
        if (act[j]) {
          const int64_t src = base + (int64_t)p * row_bytes;
          qk[j] = *(const kv_u32x4*)(kbase + src);
          if (vbase) qv[j] = *(const kv_u32x4*)(vbase + src);
        }
      }
    }
    __syncthreads();  // the whole chunk is read before any of it is written
#pragma unroll
    for (int j = 0; j < kKvPerLane; ++j) {
      if (act[j]) {
        *(kv_u32x4*)(kbase + dst[j]) = qk[j];
        if (vbase) *(kv_u32x4*)(vbase + dst[j]) = qv[j];
      }
    }
    __syncthreads();
  }
}

}  // namespace
}  // namespace sv

namespace {

// Checks shared by both entry points, then the launch.
sv_status_t kv_launch(sv::KvArgs a, int32_t elem_bytes, int32_t L, int32_t B, int32_t H, int32_t S, int32_t D,
                      int32_t P, bool layers, void* stream) {
  if (!a.root || !a.path || !a.path_len || !a.cache_len) return SV_ERR_NULL_ARG;
  if (L < 0 || B < 0 || H < 0 || S < 1 || D < 1 || P < 1 || P > sv::kKvMaxPath) return SV_ERR_BAD_SHAPE;
  if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4) return SV_ERR_BAD_DTYPE;
  // Rows move as 16-byte vectors: a row is a whole number of them.
  const int64_t row_bytes = (int64_t)D * elem_bytes;
  if (row_bytes % 16 != 0 || row_bytes > sv::kKvMaxRowBytes) return SV_ERR_BAD_SHAPE;
  const int64_t groups = (int64_t)L * B;
  if (groups >= (1ll << 31) || (int64_t)H * P * (row_bytes / 16) >= (1ll << 31)) return SV_ERR_BAD_SHAPE;
  if (groups == 0 || H == 0) return SV_OK;
  a.B = B;
  a.H = H;
  a.S = S;
  a.vpr = (int32_t)(row_bytes / 16);
  a.P = P;
  const dim3 grid((unsigned)groups), block(sv::kKvThreads);
  if (layers)
    hipLaunchKernelGGL(sv::kv_rollback_kernel<true>, grid, block, P * sizeof(int32_t), (hipStream_t)stream, a);
  else
    hipLaunchKernelGGL(sv::kv_rollback_kernel<false>, grid, block, P * sizeof(int32_t), (hipStream_t)stream, a);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}

}  // namespace

extern "C" {

sv_status_t sv_kv_rollback(void* k_cache, void* v_cache, int32_t elem_bytes, int32_t L, int32_t B, int32_t H,
                           int32_t S, int32_t D, const int32_t* root_pos, const int32_t* path, int32_t P,
                           const int32_t* path_len, int32_t* cache_len, void* stream) {
  if (!k_cache) return SV_ERR_NULL_ARG;
  // The caches are 16-byte aligned.
  if ((uintptr_t)k_cache % 16 != 0 || (uintptr_t)v_cache % 16 != 0) return SV_ERR_BAD_ARG;
  sv::KvArgs a = {};
  a.k = (uint8_t*)k_cache;
  a.v = (uint8_t*)v_cache;
  a.root = root_pos;
  a.path = path;
  a.path_len = path_len;
  a.cache_len = cache_len;
  return kv_launch(a, elem_bytes, L, B, H, S, D, P, false, stream);
}

sv_status_t sv_kv_rollback_layers(void* const* k_layers, void* const* v_layers, int32_t elem_bytes, int32_t L,
                                  int32_t B, int32_t H, int32_t S, int32_t D, const int32_t* root_pos,
                                  const int32_t* path, int32_t P, const int32_t* path_len, int32_t* cache_len,
                                  void* stream) {
  if (!k_layers) return SV_ERR_NULL_ARG;
  sv::KvArgs a = {};
  a.k_layers = (const uint64_t*)k_layers;
  a.v_layers = (const uint64_t*)v_layers;
  a.root = root_pos;
  a.path = path;
  a.path_len = path_len;
  a.cache_len = cache_len;
  return kv_launch(a, elem_bytes, L, B, H, S, D, P, true, stream);
}

}  // extern "C"
