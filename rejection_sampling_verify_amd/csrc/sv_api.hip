// sv_api.hip — the C ABI of include/spec_verify.h: argument validation,
// workspace layout, launch configuration. Host code only.
#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstring>

#include "../../include/spec_verify.h"
#include "sv_device.h"
#include "sv_internal.h"

namespace sv {

static size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int32_t max_chunks(int32_t V) {
  // Smallest chunk: one fp32 vector per thread.
  const int32_t smallest = kThreads * 4;
  return (V + smallest - 1) / smallest;
}

WsLayout ws_layout(int32_t B, int32_t rows, int32_t nchunks) {
  WsLayout L;
  size_t off = 0;
  L.done = off;
  off += 256;
  L.seq = off;
  off = round_up(off + (size_t)B * sizeof(SeqState), 256);
  L.p1 = off;
  off = round_up(off + (size_t)B * rows * nchunks * sizeof(P1Slot), 256);
  L.p2 = off;
  off = round_up(off + (size_t)B * nchunks * sizeof(P2Slot), 256);
  L.tree_slot = off;
  off = round_up(off + (size_t)B * rows * nchunks * sizeof(TreeSlot), 256);
  L.work = off;
  off = round_up(off + (size_t)B * sizeof(WorkRec), 256);
  L.total = off;
  return L;
}

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];
std::atomic<int> g_occ[kMaxDevices][12];
std::atomic<int> g_tree_occ[kMaxDevices][4];

struct Tiling {
  int kv, chunk, nchunks;
};

// Pass-1 items a launch should hold at least (one per CU), so that small
// batches still spread over the whole GPU. Above that, longer chunks win: at
// chain_bf16_peaked (640 row reads of 32000) chunks of eight vectors per
// thread (1280 items, one resident wave of them) take 31.7 us a call against
// 36.9 us for two vectors per thread (5120 items).
constexpr long long kTargetItems = 256;

// Chunk length: as long as possible (8 vectors per thread) while the pass-1
// item count stays at or above the target. forced_kv (a power of two up to 8)
// fixes the vectors per thread instead; 0 picks them.
Tiling pick_tiling(long long rows, int32_t V, bool bf16, int forced_kv = 0) {
  const int ev = bf16 ? 8 : 4;
  int kv = kMaxVecsPerThread;
  if (forced_kv >= 1 && forced_kv <= kMaxVecsPerThread && (forced_kv & (forced_kv - 1)) == 0) {
    kv = forced_kv;
  } else {
    while (kv > 1) {
      const long long chunk = (long long)kThreads * ev * kv;
      const long long items = rows * ((V + chunk - 1) / chunk);
      if (items >= kTargetItems) break;
      kv >>= 1;
    }
  }
  Tiling t;
  t.kv = kv;
  t.chunk = kThreads * ev * kv;
  t.nchunks = (V + t.chunk - 1) / t.chunk;
  return t;
}

bool device_info(int* dev, int* cus) {
  if (hipGetDevice(dev) != hipSuccess || *dev < 0 || *dev >= kMaxDevices) return false;
  int n = g_cus[*dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, *dev) != hipSuccess || n <= 0)
      return false;
    g_cus[*dev].store(n, std::memory_order_relaxed);
  }
  *cus = n;
  return true;
}

// Resident workgroups per CU of the pass-2 launch, queried once per device
// and configuration.
int p2_occupancy(int dev, bool bf16, bool vec) {
  const int k = 4 + (bf16 ? 2 : 0) + (vec ? 1 : 0);
  int n = g_occ[dev][k].load(std::memory_order_relaxed);
  if (n <= 0) {
    n = chain_p2_occupancy(bf16, vec);
    if (n <= 0) n = 1;
    g_occ[dev][k].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Resident workgroups per CU of the sampled-tree walk launch.
int tree_walk_occupancy_cached(int dev, bool bf16, bool vec) {
  const int k = 8 + (bf16 ? 2 : 0) + (vec ? 1 : 0);
  int n = g_occ[dev][k].load(std::memory_order_relaxed);
  if (n <= 0) {
    n = tree_sample_walk_occupancy(bf16, vec);
    if (n <= 0) n = 1;
    g_occ[dev][k].store(n, std::memory_order_relaxed);
  }
  return n;
}

int tree_occupancy_cached(int dev, bool bf16, bool vec) {
  const int k = (bf16 ? 2 : 0) + (vec ? 1 : 0);
  int n = g_tree_occ[dev][k].load(std::memory_order_relaxed);
  if (n <= 0) {
    n = tree_occupancy(bf16, vec);
    if (n <= 0) n = 1;
    g_tree_occ[dev][k].store(n, std::memory_order_relaxed);
  }
  return n;
}

// The raw value of an enum argument: callers through the C ABI may pass any
// int, and a C++ load of an enum value outside its listed range is undefined,
// so it is validated as an int.
template <typename E>
int raw_value(const E& e) {
  int v;
  static_assert(sizeof(E) == sizeof(int), "enum arguments are int-sized");
  std::memcpy(&v, &e, sizeof(v));
  return v;
}

bool dtype_ok(int dt) { return dt == SV_DTYPE_F32 || dt == SV_DTYPE_BF16; }

bool aligned16(const void* p, int64_t stride_bytes) {
  return ((uintptr_t)p % 16 == 0) && (stride_bytes % 16 == 0);
}

sv_status_t check_workspace(void* ws, size_t bytes, size_t need) {
  if (ws == nullptr || bytes < need) return SV_ERR_WORKSPACE;
  if ((uintptr_t)ws % 256 != 0) return SV_ERR_BAD_ARG;
  return SV_OK;
}

// Host-side validation of the chain entry points' arguments (no HIP call).
sv_status_t check_chain_args(const void* target, int64_t t_stride, const void* draft, int64_t d_stride,
                             int dtype, const int32_t* ids, int32_t B, int32_t gamma, int32_t V,
                             uint64_t offset, uint32_t seq_base, const int32_t* out_tokens, const int32_t* out_n) {
  if (!target || !ids || !out_tokens || !out_n) return SV_ERR_NULL_ARG;
  if (B < 0 || B > SV_MAX_BATCH || gamma < 1 || gamma > SV_MAX_GAMMA || V < 1 || V > (1 << 30))
    return SV_ERR_BAD_SHAPE;
  if (!dtype_ok(dtype)) return SV_ERR_BAD_DTYPE;
  if (t_stride < V || (draft && d_stride < V)) return SV_ERR_BAD_ARG;
  if (offset >= (1ull << 31)) return SV_ERR_BAD_ARG;
  if ((uint64_t)seq_base + (uint64_t)B > (1ull << 32)) return SV_ERR_BAD_ARG;
  return SV_OK;
}

// forced_kv, forced_p2: the debug entry point's fixed tiling (0: chosen here).
sv_status_t run_chain(const void* target, int64_t t_stride, const void* draft, int64_t d_stride,
                      int dtype, const int32_t* ids, const float* temperature, int32_t B,
                      int32_t gamma, int32_t V, uint64_t seed, uint64_t offset, uint32_t seq_base,
                      int32_t* out_tokens, int32_t* out_n, const sv_diag_t* diag, void* workspace,
                      size_t workspace_bytes, void* stream, int forced_kv = 0, int forced_p2 = 0,
                      bool clear_workspace = false) {
  const sv_status_t args_ok =
      check_chain_args(target, t_stride, draft, d_stride, dtype, ids, B, gamma, V, offset, seq_base, out_tokens, out_n);
  if (args_ok != SV_OK) return args_ok;
  if (forced_kv < 0 || forced_p2 < 0) return SV_ERR_BAD_ARG;
  const size_t need = sv_workspace_bytes(B, gamma + 1, V);
  const sv_status_t ws_ok = check_workspace(workspace, workspace_bytes, need);
  if (ws_ok != SV_OK) return ws_ok;
  if (B == 0) return SV_OK;

  const bool bf16 = (dtype == SV_DTYPE_BF16);
  const int es = bf16 ? 2 : 4;
  const bool vec = aligned16(target, t_stride * es) && (!draft || aligned16(draft, d_stride * es));
  const Tiling tl = pick_tiling((long long)B * gamma * (draft ? 2 : 1), V, bf16, forced_kv);
  const WsLayout L = ws_layout(B, gamma + 1, max_chunks(V));
  uint8_t* ws = (uint8_t*)workspace;

  int dev = 0, cus = 0;
  if (!device_info(&dev, &cus)) return SV_ERR_HIP;

  ChainArgs a;
  std::memset(&a, 0, sizeof(a));
  a.target = (const uint8_t*)target;
  a.t_stride = t_stride * es;
  a.draft = (const uint8_t*)draft;
  a.d_stride = d_stride * es;
  a.d_rows = gamma;
  a.ids = ids;
  a.temperature = temperature;
  a.B = B;
  a.gamma = gamma;
  a.V = V;
  a.chunk = tl.chunk;
  a.nchunks = tl.nchunks;
  a.kv = tl.kv;
  // Pass-2 chunks: the second launch sizes them on the device, once the
  // number of sequences with a pending draw is known, as many per row as fill
  // one resident wave of its workgroups, each at least four streaming units
  // long (one unit: one vector per thread).
  {
    const int unit = kThreads * (bf16 ? 8 : 4);
    const long long cap = std::max<long long>(1, (V + 4 * unit - 1) / (4 * unit));
    a.p2_stride = max_chunks(V);
    a.p2_unit = unit;
    // A forced count may cut rows down to one unit per chunk.
    const long long cap1 = (V + unit - 1) / unit;
    a.p2_force = forced_p2 > 0 ? (int32_t)std::min<long long>(forced_p2, cap1) : 0;
    a.p2_cap = a.p2_force > 0 ? a.p2_force : (int32_t)cap;
    // At most kP2Resident per CU even where more would fit: seven per CU
    // measured no faster at either large chain workload.
    const long long resident2 = (long long)cus * std::min(kP2Resident, p2_occupancy(dev, bf16, vec));
    // No more workgroups than the draws can use (B rows of at most cap
    // chunks): a small batch launches only those.
    const long long grid2 = a.p2_force > 0 ? (long long)B * a.p2_force
                                           : std::max<long long>(B, std::min<long long>(resident2, (long long)B * cap));
    if (grid2 >= (1ll << 31)) return SV_ERR_BAD_SHAPE;
    a.p2_grid = (int32_t)grid2;
  }
  a.key0 = (uint32_t)seed;
  a.key1 = (uint32_t)(seed >> 32);
  a.ctr_accept = (uint32_t)(2u * (uint32_t)offset);
  a.ctr_noise = (uint32_t)(2u * (uint32_t)offset + 1u);
  a.seq_base = seq_base;
  a.out_tokens = out_tokens;
  a.out_n = out_n;
  if (diag) {
    a.d_accept = diag->accept_prob;
    a.d_logzt = diag->logz_target;
    a.d_logzd = diag->logz_draft;
    a.d_beta = diag->residual_mass;
  }
  a.done = (uint32_t*)(ws + L.done);
  a.seq = (SeqState*)(ws + L.seq);
  a.p1 = (P1Slot*)(ws + L.p1);
  a.p2 = (P2Slot*)(ws + L.p2);
  a.work = (WorkRec*)(ws + L.work);
  a.spin_limit = 1u << 22;
  const long long n1 = (long long)gamma * tl.nchunks * (draft ? 2 : 1);
  if ((long long)B * (n1 + 1) >= (1ll << 31)) return SV_ERR_BAD_SHAPE;

  // Two launches: pass 1 over every (sequence, position, chunk) followed by
  // the decisions, then pass 2.
  hipStream_t s = (hipStream_t)stream;
  // The allocation-free variant's scratch keeps the last call's contents:
  // the range this call uses is zeroed first (a fill kernel).
  if (clear_workspace && launch_fill_zero(workspace, need, s) != hipSuccess) return SV_ERR_HIP;
  if (launch_chain_p1(a, bf16, vec, s) != hipSuccess) return SV_ERR_HIP;
  if (launch_chain_p2(a, bf16, vec, s) != hipSuccess) return SV_ERR_HIP;
  return SV_OK;
}

// Scratch memory of the allocation-free entry point: a file-scope device
// array, one copy per GPU, held until the process ends. Host code never uses
// the array's name as an address (on the host it is only a stand-in for the
// symbol): the device address comes from hipGetSymbolAddress, looked up once
// per device with that device current and kept here.
constexpr size_t kScratchBytes = SV_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) uint8_t scratch[kScratchBytes];
std::atomic<void*> g_scratch[kMaxDevices];

void* scratch_address(int dev) {
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace
}  // namespace sv

extern "C" {

size_t sv_workspace_bytes(int32_t B, int32_t rows, int32_t V) {
  if (B < 0 || B > SV_MAX_BATCH || rows < 1 || rows > SV_MAX_TREE_NODES || V < 1 || V > (1 << 30)) return 0;
  return sv::ws_layout(B, rows, sv::max_chunks(V)).total;
}

sv_status_t sv_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
  if (workspace == nullptr) return SV_ERR_NULL_ARG;
  if ((uintptr_t)workspace % 256 != 0 || workspace_bytes % 4 != 0) return SV_ERR_BAD_ARG;
  return sv::launch_fill_zero(workspace, workspace_bytes, (hipStream_t)stream) == hipSuccess ? SV_OK : SV_ERR_HIP;
}

const char* sv_status_string(sv_status_t status) {
  // Callers through the C ABI may pass any int: the code is read as the raw
  // value (a C++ load of an enum outside its listed range is undefined).
  int code;
  std::memcpy(&code, &status, sizeof(code));
  switch (code) {
    case SV_OK: return "success";
    case SV_ERR_NULL_ARG: return "a required pointer is NULL";
    case SV_ERR_BAD_SHAPE: return "batch, draft length, node count, vocabulary or depth out of range";
    case SV_ERR_BAD_DTYPE: return "unknown logits dtype";
    case SV_ERR_BAD_ARG: return "bad stride, offset or alignment";
    case SV_ERR_WORKSPACE: return "workspace missing or too small";
    case SV_ERR_HIP: return "HIP runtime or launch failure";
    case SV_ERR_SCRATCH_LIMIT: return "call needs more than the allocation-free entry point's scratch memory";
  }
  return "unknown status";
}

sv_status_t spec_verify_sample(const void* target_logits, int64_t target_row_stride, const void* draft_logits,
                               int64_t draft_row_stride, sv_dtype_t dtype, const int32_t* draft_ids,
                               const float* temperature, int32_t B, int32_t gamma, int32_t V, uint64_t seed,
                               uint64_t offset, uint32_t seq_base, int32_t* out_tokens, int32_t* out_num_accepted,
                               const sv_diag_t* diag, void* workspace, size_t workspace_bytes, void* stream) {
  if (!temperature) return SV_ERR_NULL_ARG;
  return sv::run_chain(target_logits, target_row_stride, draft_logits, draft_row_stride, sv::raw_value(dtype), draft_ids,
                       temperature, B, gamma, V, seed, offset, seq_base, out_tokens, out_num_accepted, diag,
                       workspace, workspace_bytes, stream);
}

sv_status_t sv_debug_sample_tiled(const void* target_logits, int64_t target_row_stride, const void* draft_logits,
                                  int64_t draft_row_stride, sv_dtype_t dtype, const int32_t* draft_ids,
                                  const float* temperature, int32_t B, int32_t gamma, int32_t V, uint64_t seed,
                                  uint64_t offset, uint32_t seq_base, int32_t* out_tokens,
                                  int32_t* out_num_accepted, const sv_diag_t* diag, void* workspace,
                                  size_t workspace_bytes, void* stream, int32_t p1_vectors, int32_t p2_chunks) {
  if (!temperature) return SV_ERR_NULL_ARG;
  if (p1_vectors < 0 || p1_vectors > sv::kMaxVecsPerThread || (p1_vectors & (p1_vectors - 1)) != 0 ||
      p2_chunks < 0)
    return SV_ERR_BAD_ARG;
  return sv::run_chain(target_logits, target_row_stride, draft_logits, draft_row_stride, sv::raw_value(dtype), draft_ids,
                       temperature, B, gamma, V, seed, offset, seq_base, out_tokens, out_num_accepted, diag,
                       workspace, workspace_bytes, stream, p1_vectors, p2_chunks);
}

sv_status_t spec_verify_sample_noalloc(const void* target_logits, int64_t target_row_stride,
                                       const void* draft_logits, int64_t draft_row_stride, sv_dtype_t dtype,
                                       const int32_t* draft_ids, const float* temperature, int32_t B,
                                       int32_t gamma, int32_t V, uint64_t seed, uint64_t offset,
                                       uint32_t seq_base, int32_t* out_tokens, int32_t* out_num_accepted,
                                       const sv_diag_t* diag, void* stream) {
  if (!temperature) return SV_ERR_NULL_ARG;
  const sv_status_t args_ok = sv::check_chain_args(target_logits, target_row_stride, draft_logits, draft_row_stride,
                                                   sv::raw_value(dtype), draft_ids, B, gamma, V, offset, seq_base, out_tokens,
                                                   out_num_accepted);
  if (args_ok != SV_OK) return args_ok;
  const size_t need = sv_workspace_bytes(B, gamma + 1, V);
  if (need > sv::kScratchBytes) return SV_ERR_SCRATCH_LIMIT;
  if (B == 0) return SV_OK;
  int dev = 0, cus = 0;
  if (!sv::device_info(&dev, &cus)) return SV_ERR_HIP;
  void* ws = sv::scratch_address(dev);
  if (ws == nullptr) return SV_ERR_HIP;
  return sv::run_chain(target_logits, target_row_stride, draft_logits, draft_row_stride, sv::raw_value(dtype), draft_ids,
                       temperature, B, gamma, V, seed, offset, seq_base, out_tokens, out_num_accepted, diag, ws,
                       need, stream, 0, 0, /*clear_workspace=*/true);
}

sv_status_t spec_verify_greedy(const void* target_logits, int64_t target_row_stride, sv_dtype_t dtype,
                               const int32_t* draft_ids, int32_t B, int32_t gamma, int32_t V, int32_t* out_tokens,
                               int32_t* out_num_accepted, void* workspace, size_t workspace_bytes, void* stream) {
  return sv::run_chain(target_logits, target_row_stride, nullptr, 0, sv::raw_value(dtype), draft_ids, nullptr, B, gamma,
                       V, 0, 0, 0,
                       out_tokens, out_num_accepted, nullptr, workspace, workspace_bytes, stream);
}

sv_status_t spec_verify_tree(const void* target_logits, int64_t target_row_stride, sv_dtype_t dtype,
                             const int32_t* parents, const int32_t* depth, const int32_t* node_tokens, int32_t B,
                             int32_t N, int32_t V, int32_t max_depth, int32_t* out_path, int32_t* out_path_len,
                             int32_t* out_bonus, void* workspace, size_t workspace_bytes, void* stream) {
  if (!target_logits || !parents || !depth || !node_tokens || !out_path || !out_path_len || !out_bonus)
    return SV_ERR_NULL_ARG;
  if (B < 0 || B > SV_MAX_BATCH || N < 1 || N > SV_MAX_TREE_NODES || V < 1 || V > (1 << 30) || max_depth < 0 ||
      max_depth >= N)
    return SV_ERR_BAD_SHAPE;
  if (!sv::dtype_ok(sv::raw_value(dtype))) return SV_ERR_BAD_DTYPE;
  if (target_row_stride < V) return SV_ERR_BAD_ARG;
  const size_t need = sv_workspace_bytes(B, N, V);
  const sv_status_t ws_ok = sv::check_workspace(workspace, workspace_bytes, need);
  if (ws_ok != SV_OK) return ws_ok;
  if (B == 0) return SV_OK;
  const bool bf16 = (dtype == SV_DTYPE_BF16);
  const int es = bf16 ? 2 : 4;
  const sv::Tiling tl = sv::pick_tiling((long long)B * N, V, bf16);
  if ((long long)B * N * tl.nchunks + B >= (1ll << 31)) return SV_ERR_BAD_SHAPE;
  const sv::WsLayout L = sv::ws_layout(B, N, sv::max_chunks(V));
  uint8_t* ws = (uint8_t*)workspace;
  sv::TreeArgs a;
  std::memset(&a, 0, sizeof(a));
  a.target = (const uint8_t*)target_logits;
  a.t_stride = target_row_stride * es;
  a.parents = parents;
  a.depth = depth;
  a.tokens = node_tokens;
  a.B = B;
  a.N = N;
  a.V = V;
  a.max_depth = max_depth;
  a.chunk = tl.chunk;
  a.nchunks = tl.nchunks;
  a.kv = tl.kv;
  a.out_path = out_path;
  a.out_path_len = out_path_len;
  a.out_bonus = out_bonus;
  a.done = (uint32_t*)(ws + L.done);
  a.slot = (sv::TreeSlot*)(ws + L.tree_slot);
  const bool vec = sv::aligned16(target_logits, a.t_stride);
  a.spin_limit = 1u << 22;
  int dev = 0, cus = 0;
  if (!sv::device_info(&dev, &cus)) return SV_ERR_HIP;
  // Lag: about one resident GPU's worth of items between a sequence's items
  // and its decision.
  const long long n1 = (long long)N * tl.nchunks;
  const long long resident = (long long)cus * sv::tree_occupancy_cached(dev, bf16, vec);
  a.lag = (int32_t)std::min<long long>((resident + n1 - 1) / n1 + 1, 1 << 20);
  return sv::launch_tree(a, bf16, vec, (hipStream_t)stream) == hipSuccess ? SV_OK : SV_ERR_HIP;
}

static_assert(SV_MAX_TREE_NODES == sv::kMaxTreeNodes, "LDS copies of a tree hold SV_MAX_TREE_NODES nodes");

sv_status_t spec_verify_tree_sample(const void* target_logits, int64_t target_row_stride, const void* draft_logits,
                                    int64_t draft_row_stride, sv_dtype_t dtype, const int32_t* parents,
                                    const int32_t* depth, const int32_t* node_tokens, const float* temperature,
                                    int32_t B, int32_t N, int32_t V, int32_t max_depth, uint64_t seed,
                                    uint64_t offset, uint32_t seq_base, int32_t siblings_without_replacement,
                                    int32_t* out_path,
                                    int32_t* out_path_len, int32_t* out_token, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  if (!target_logits || !draft_logits || !parents || !depth || !node_tokens || !temperature || !out_path ||
      !out_path_len || !out_token)
    return SV_ERR_NULL_ARG;
  if (B < 0 || B > SV_MAX_BATCH || N < 1 || N > SV_MAX_TREE_NODES || V < 1 || V > (1 << 30) || max_depth < 0 ||
      max_depth >= N)
    return SV_ERR_BAD_SHAPE;
  if (!sv::dtype_ok(sv::raw_value(dtype))) return SV_ERR_BAD_DTYPE;
  if (target_row_stride < V || draft_row_stride < V) return SV_ERR_BAD_ARG;
  if (offset >= (1ull << 31)) return SV_ERR_BAD_ARG;
  if (siblings_without_replacement != 0 && siblings_without_replacement != 1) return SV_ERR_BAD_ARG;
  if ((uint64_t)seq_base + (uint64_t)B > (1ull << 32)) return SV_ERR_BAD_ARG;
  const size_t need = sv_workspace_bytes(B, N, V);
  const sv_status_t ws_ok = sv::check_workspace(workspace, workspace_bytes, need);
  if (ws_ok != SV_OK) return ws_ok;
  if (B == 0) return SV_OK;
  const bool bf16 = (dtype == SV_DTYPE_BF16);
  const int es = bf16 ? 2 : 4;
  const sv::Tiling tl = sv::pick_tiling((long long)B * N * 2, V, bf16);
  if ((long long)B * N * 2 * tl.nchunks >= (1ll << 31)) return SV_ERR_BAD_SHAPE;
  const sv::WsLayout L = sv::ws_layout(B, N, sv::max_chunks(V));
  uint8_t* ws = (uint8_t*)workspace;
  int dev = 0, cus = 0;
  if (!sv::device_info(&dev, &cus)) return SV_ERR_HIP;

  sv::TreeSampleArgs a;
  std::memset(&a, 0, sizeof(a));
  sv::ChainArgs& c = a.c;
  c.target = (const uint8_t*)target_logits;
  c.t_stride = target_row_stride * es;
  c.draft = (const uint8_t*)draft_logits;
  c.d_stride = draft_row_stride * es;
  c.d_rows = N;
  c.temperature = temperature;
  c.B = B;
  c.gamma = N - 1;  // target row (b, v) is row b * N + v
  c.V = V;
  c.chunk = tl.chunk;
  c.nchunks = tl.nchunks;
  c.kv = tl.kv;
  c.p2_stride = sv::max_chunks(V);
  c.key0 = (uint32_t)seed;
  c.key1 = (uint32_t)(seed >> 32);
  c.ctr_accept = (uint32_t)(2u * (uint32_t)offset);
  c.ctr_noise = (uint32_t)(2u * (uint32_t)offset + 1u);
  c.seq_base = seq_base;
  c.done = (uint32_t*)(ws + L.done);
  c.seq = (sv::SeqState*)(ws + L.seq);
  c.p1 = (sv::P1Slot*)(ws + L.p1);
  c.p2 = (sv::P2Slot*)(ws + L.p2);
  c.spin_limit = 1u << 22;
  a.parents = parents;
  a.depth = depth;
  a.tokens = node_tokens;
  a.N = N;
  a.max_depth = max_depth;
  // The walk's second buffer of workgroup parts: the greedy tree's slots,
  // unused here (B * N * nchunks 8-byte slots hold B * nchunks 16-byte parts
  // for N >= 2; a one-node tree never needs the second buffer).
  a.slot2 = (sv::P2Slot*)(ws + L.tree_slot);
  a.wor = siblings_without_replacement;
  a.out_path = out_path;
  a.out_len = out_path_len;
  a.out_token = out_token;
  const bool vec = sv::aligned16(target_logits, c.t_stride) && sv::aligned16(draft_logits, c.d_stride);
  // Walk: about 8K elements of a row per workgroup (whole streaming rounds),
  // and as many sequences per launch as keep every workgroup resident.
  const int unit = sv::kThreads * (bf16 ? 8 : 4);
  const int per_wg = std::max(unit, 8192);
  const int w0 = std::max(1, (V + per_wg - 1) / per_wg);
  a.wlen = ((V + w0 - 1) / w0 + unit - 1) / unit * unit;
  // At most 256 workgroups per sequence (each stages the parts, one per thread).
  const int min_wlen = ((V + 255) / 256 + unit - 1) / unit * unit;
  a.wlen = std::max(a.wlen, min_wlen);
  a.W = (V + a.wlen - 1) / a.wlen;
  if (a.W > c.p2_stride) return SV_ERR_BAD_SHAPE;
  const long long resident = (long long)cus * sv::tree_walk_occupancy_cached(dev, bf16, vec);
  if (a.W > resident) return SV_ERR_BAD_SHAPE;
  const long long per_launch = std::max<long long>(1, resident / a.W);
  hipStream_t st = (hipStream_t)stream;
  for (long long b0 = 0; b0 < B; b0 += per_launch) {
    a.b_base = (int32_t)b0;
    a.b_count = (int32_t)std::min<long long>(per_launch, B - b0);
    if (sv::launch_tree_sample_walk(a, bf16, vec, st) != hipSuccess) return SV_ERR_HIP;
  }
  return SV_OK;
}

}  // extern "C"
